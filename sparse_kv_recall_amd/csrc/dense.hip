// Dense layers of the weight-bearing decode step: one token (batch 1) through a
// Qwen3-family decoder layer (RMSNorm, fused q/k/v projection with per-head q/k norm
// and rotary positions, output projection, gated-SiLU MLP), plus embedding lookup,
// final norm and the step select.
//
// Why these run here: an On-Demand-Attention step that recalls recomputes the whole
// model for the current token (On-Demand Attention summary page, "Approach"), and the
// recall head reads the Local pass's final hidden state, so the dense layers sit on
// the decode path next to the attention kernels.
//
// How (gfx950): batch-1 projections are GEMVs bound by reading the bf16 weights once,
// so there is no MFMA here (a matrix core would see one useful column). Each wave owns
// whole rows: its lanes issue all 16-byte weight loads of its rows first, then the
// workgroup stages the transformed input vector in LDS (RMSNorm or SwiGLU prologue),
// then every lane forms partial dot products that a DPP wave reduction sums in a fixed
// order (deterministic). The residual add is fused into the store. The q/k/v kernel
// gives one workgroup to each head, so the head's RMS norm and the rotary pairing
// (i, i + 64) stay inside the workgroup; rotary angles are computed in fp64.
#include <math.h>

#include "sk_internal.h"

namespace sk {
namespace {

constexpr int kGemvWaves = 4;   // waves per GEMV workgroup
constexpr int kQkvThreads = 1024;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Sum over the 64 lanes, the same value in every lane: swap neighbours, swap pairs,
// rotate rows by 4 and 8 (DPP), then the four row sums in a fixed order.
__device__ inline float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Sum of v over the workgroup (fixed order); `red` holds one float per wave.
__device__ inline float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < nw; ++w) s += red[w];
  __syncthreads();
  return s;
}

__device__ inline bool gated_off(const int32_t* sel, int sel_value) { return sel && sel[0] != sel_value; }

// Dot product of one 8-element weight chunk (bf16) with 8 floats of x in LDS.
__device__ inline float dot8(u32x4 w, const float* xs) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(xs);
  const f32x4 b = *reinterpret_cast<const f32x4*>(xs + 4);
  float s = 0.f;
  s = fmaf(__uint_as_float(w.x << 16), a.x, s);
  s = fmaf(__uint_as_float(w.x & 0xFFFF0000u), a.y, s);
  s = fmaf(__uint_as_float(w.y << 16), a.z, s);
  s = fmaf(__uint_as_float(w.y & 0xFFFF0000u), a.w, s);
  s = fmaf(__uint_as_float(w.z << 16), b.x, s);
  s = fmaf(__uint_as_float(w.z & 0xFFFF0000u), b.y, s);
  s = fmaf(__uint_as_float(w.w << 16), b.z, s);
  s = fmaf(__uint_as_float(w.w & 0xFFFF0000u), b.w, s);
  return s;
}

// Stage the prologue's input vector (cols floats) in LDS.
template <int PRO>
__device__ inline void stage_input(const float* __restrict__ x, const uint16_t* __restrict__ gamma, float eps,
                                   int cols, float* xs, float* red) {
  if (PRO == SK_PRO_RMSNORM) {
    float ss = 0.f;
    for (int i = threadIdx.x; i < cols; i += blockDim.x) {
      const float v = x[i];
      ss = fmaf(v, v, ss);
    }
    const float r = 1.f / sqrtf(block_sum(ss, red) / float(cols) + eps);
    for (int i = threadIdx.x; i < cols; i += blockDim.x) xs[i] = x[i] * r * bf16f(gamma[i]);
  } else if (PRO == SK_PRO_SWIGLU) {
    for (int i = threadIdx.x; i < cols; i += blockDim.x) {
      const float g = x[i];
      xs[i] = g / (1.f + expf(-g)) * x[cols + i];
    }
  } else {
    for (int i = threadIdx.x; i < cols; i += blockDim.x) xs[i] = x[i];
  }
  __syncthreads();
}

// RW rows per wave, J 16-byte chunks per lane per row (cols = 512 J).
template <int J, int RW, int PRO>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_kernel(const uint16_t* __restrict__ W, int rows, int cols,
                                                               const float* __restrict__ x,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               const float* residual, float* y, const int32_t* sel,
                                                               int sel_value) {
  if (gated_off(sel, sel_value)) return;
  extern __shared__ float xs[];
  __shared__ float red[kGemvWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = (blockIdx.x * kGemvWaves + wave) * RW;
  u32x4 w[RW][J];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const u32x4* row = reinterpret_cast<const u32x4*>(W + size_t(min(r0 + r, rows - 1)) * cols);
#pragma unroll
    for (int j = 0; j < J; ++j) w[r][j] = __builtin_nontemporal_load(row + lane + 64 * j);
  }
  stage_input<PRO>(x, gamma, eps, cols, xs, red);
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) acc += dot8(w[r][j], xs + 8 * (lane + 64 * j));
    acc = wave_sum(acc);
    if (lane == 0 && r0 + r < rows) y[r0 + r] = acc + (residual ? residual[r0 + r] : 0.f);
  }
}

// One workgroup per head (q heads, then k heads, then v heads); 16 waves, 8 rows each,
// RB rows in flight per wave at a time.
template <int J>
__global__ __launch_bounds__(kQkvThreads) void qkv_kernel(const uint16_t* __restrict__ W, const float* __restrict__ h,
                                                          const uint16_t* __restrict__ g_attn,
                                                          const uint16_t* __restrict__ g_q,
                                                          const uint16_t* __restrict__ g_k, int hidden, int Hq,
                                                          int Hkv, float eps, float rope_base,
                                                          const int32_t* __restrict__ seq_lens, float* q_out,
                                                          uint16_t* k_out, uint16_t* v_out, const int32_t* sel,
                                                          int sel_value) {
  constexpr int RB = (J <= 2) ? 8 : (J <= 4 ? 4 : (J <= 8 ? 2 : 1));
  if (gated_off(sel, sel_value)) return;
  extern __shared__ float xs[];
  __shared__ float red[kQkvThreads / 64];
  __shared__ float s_val[kHeadDim];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head = blockIdx.x;
  const uint16_t* Wh = W + size_t(head) * kHeadDim * hidden;
  u32x4 w[RB][J];
  auto load_rows = [&](int rb) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const u32x4* row = reinterpret_cast<const u32x4*>(Wh + size_t(8 * wave + rb + r) * hidden);
#pragma unroll
      for (int j = 0; j < J; ++j) w[r][j] = __builtin_nontemporal_load(row + lane + 64 * j);
    }
  };
  load_rows(0);
  stage_input<SK_PRO_RMSNORM>(h, g_attn, eps, hidden, xs, red);
  for (int rb = 0; rb < 8; rb += RB) {
    if (rb > 0) load_rows(rb);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) acc += dot8(w[r][j], xs + 8 * (lane + 64 * j));
      acc = wave_sum(acc);
      if (lane == 0) s_val[8 * wave + rb + r] = acc;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  const bool is_q = head < Hq, is_v = head >= Hq + Hkv;
  float v = (t < kHeadDim) ? s_val[t] : 0.f;
  // per-head RMS norm of q and k (sum over the 128 values, fixed order)
  const float ss = block_sum(v * v, red);
  if (!is_v && t < kHeadDim) {
    const uint16_t* g = is_q ? g_q : g_k;
    v = v * (1.f / sqrtf(ss / float(kHeadDim) + eps)) * bf16f(g[t]);
  }
  __syncthreads();
  if (t < kHeadDim) s_val[t] = v;
  __syncthreads();
  if (t < kHeadDim) {
    float o = v;
    if (!is_v) {
      const int i = t & 63;
      const double ang = double(seq_lens[0] - 1) * pow(double(rope_base), -double(i) / 64.0);
      const float c = float(cos(ang)), s = float(sin(ang));
      o = (t < 64) ? v * c - s_val[t + 64] * s : v * c + s_val[t - 64] * s;
    }
    if (is_q) {
      q_out[head * kHeadDim + t] = o;
    } else {
      uint16_t* dst = is_v ? v_out + (head - Hq - Hkv) * kHeadDim : k_out + (head - Hq) * kHeadDim;
      dst[t] = __builtin_bit_cast(uint16_t, __bf16(o));
    }
  }
}

__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                       int dim, float eps, float* out, const int32_t* sel,
                                                       int sel_value) {
  __shared__ float red[16];
  if (gated_off(sel, sel_value)) return;
  float ss = 0.f;
  for (int i = threadIdx.x; i < dim; i += blockDim.x) ss = fmaf(x[i], x[i], ss);
  const float r = 1.f / sqrtf(block_sum(ss, red) / float(dim) + eps);
  for (int i = threadIdx.x; i < dim; i += blockDim.x) out[i] = x[i] * r * bf16f(gamma[i]);
}

__global__ void embed_kernel(const uint16_t* __restrict__ table, int vocab, int hidden,
                             const int32_t* __restrict__ token, float* out, float* out2, const int32_t* sel,
                             int sel_value) {
  if (gated_off(sel, sel_value)) return;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= hidden) return;
  const int tok = token[0];
  const float v = (tok >= 0 && tok < vocab) ? bf16f(table[size_t(tok) * hidden + i]) : 0.f;
  out[i] = v;
  if (out2) out2[i] = v;
}

__global__ void select_kernel(const int32_t* __restrict__ gate, int gate_value, const float* __restrict__ a,
                              const float* __restrict__ b, int dim, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < dim) out[i] = (gate[0] == gate_value) ? a[i] : b[i];
}

template <int J, int RW>
int launch_gemv_j(const uint16_t* W, int rows, int cols, const float* x, int pro, const uint16_t* gamma, float eps,
                  const float* residual, float* y, const int32_t* sel, int sel_value, hipStream_t stream) {
  const int per_wg = kGemvWaves * RW;
  const dim3 grid(unsigned((rows + per_wg - 1) / per_wg)), block(64 * kGemvWaves);
  const size_t lds = size_t(cols) * 4;
  if (pro == SK_PRO_RMSNORM)
    hipLaunchKernelGGL((gemv_kernel<J, RW, SK_PRO_RMSNORM>), grid, block, lds, stream, W, rows, cols, x, gamma, eps,
                       residual, y, sel, sel_value);
  else if (pro == SK_PRO_SWIGLU)
    hipLaunchKernelGGL((gemv_kernel<J, RW, SK_PRO_SWIGLU>), grid, block, lds, stream, W, rows, cols, x, gamma, eps,
                       residual, y, sel, sel_value);
  else
    hipLaunchKernelGGL((gemv_kernel<J, RW, SK_PRO_NONE>), grid, block, lds, stream, W, rows, cols, x, gamma, eps,
                       residual, y, sel, sel_value);
  return launch_status(hipGetLastError());
}

template <int J>
int launch_qkv_j(const uint16_t* W, const float* h, const uint16_t* g_attn, const uint16_t* g_q, const uint16_t* g_k,
                 int hidden, int Hq, int Hkv, float eps, float rope_base, const int32_t* seq_lens, float* q_out,
                 uint16_t* k_out, uint16_t* v_out, const int32_t* sel, int sel_value, hipStream_t stream) {
  hipLaunchKernelGGL(qkv_kernel<J>, dim3(unsigned(Hq + 2 * Hkv)), dim3(kQkvThreads), size_t(hidden) * 4, stream, W, h,
                     g_attn, g_q, g_k, hidden, Hq, Hkv, eps, rope_base, seq_lens, q_out, k_out, v_out, sel,
                     sel_value);
  return launch_status(hipGetLastError());
}

bool valid_width(int cols) { return cols >= 512 && cols <= 16384 && cols % 512 == 0; }

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_gemv(const uint16_t* W, int32_t rows, int32_t cols, const float* x, int32_t prologue, const uint16_t* gamma,
            float eps, const float* residual, float* y, const int32_t* sel, int32_t sel_value, hipStream_t stream) {
  if (!W || !x || !y) return SK_E_NULL;
  if (prologue < SK_PRO_NONE || prologue > SK_PRO_SWIGLU || rows < 1) return SK_E_RANGE;
  if (prologue == SK_PRO_RMSNORM && !gamma) return SK_E_NULL;
  if (!valid_width(cols)) return SK_E_SHAPE;
  if (x == y) return SK_E_RANGE;
  switch (cols / 512) {
    case 1: return launch_gemv_j<1, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 2: return launch_gemv_j<2, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 3: return launch_gemv_j<3, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 4: return launch_gemv_j<4, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 6: return launch_gemv_j<6, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 8: return launch_gemv_j<8, 2>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 12: return launch_gemv_j<12, 1>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 16: return launch_gemv_j<16, 1>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 24: return launch_gemv_j<24, 1>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    case 32: return launch_gemv_j<32, 1>(W, rows, cols, x, prologue, gamma, eps, residual, y, sel, sel_value, stream);
    default: return SK_E_SHAPE;
  }
}

int sk_qkv_rope(const uint16_t* W_qkv, const float* h, const uint16_t* g_attn, const uint16_t* g_q,
                const uint16_t* g_k, int32_t hidden, int32_t q_heads, int32_t kv_heads, float eps, float rope_base,
                const int32_t* seq_lens, float* q_out, uint16_t* k_out, uint16_t* v_out, const int32_t* sel,
                int32_t sel_value, hipStream_t stream) {
  if (!W_qkv || !h || !g_attn || !g_q || !g_k || !seq_lens || !q_out || !k_out || !v_out) return SK_E_NULL;
  if (kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0) return SK_E_HEADS;
  if (q_heads + 2 * kv_heads > 65535 || !(rope_base > 0.f)) return SK_E_RANGE;
  if (!valid_width(hidden) || hidden > 4096) return SK_E_SHAPE;
  switch (hidden / 512) {
#define SK_QKV(JJ) \
  case JJ:         \
    return launch_qkv_j<JJ>(W_qkv, h, g_attn, g_q, g_k, hidden, q_heads, kv_heads, eps, rope_base, seq_lens, q_out, \
                            k_out, v_out, sel, sel_value, stream);
    SK_QKV(1)
    SK_QKV(2)
    SK_QKV(3)
    SK_QKV(4)
    SK_QKV(6)
    SK_QKV(8)
#undef SK_QKV
    default: return SK_E_SHAPE;
  }
}

int sk_rmsnorm(const float* x, const uint16_t* gamma, int32_t dim, float eps, float* out, const int32_t* sel,
               int32_t sel_value, hipStream_t stream) {
  if (!x || !gamma || !out) return SK_E_NULL;
  if (dim < 1 || dim > 16384) return SK_E_RANGE;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(1024), 0, stream, x, gamma, dim, eps, out, sel, sel_value);
  return launch_status(hipGetLastError());
}

int sk_embed(const uint16_t* table, int32_t vocab, int32_t hidden, const int32_t* token, float* out, float* out2,
             const int32_t* sel, int32_t sel_value, hipStream_t stream) {
  if (!table || !token || !out) return SK_E_NULL;
  if (vocab < 1 || hidden < 1) return SK_E_RANGE;
  hipLaunchKernelGGL(embed_kernel, dim3(unsigned((hidden + 255) / 256)), dim3(256), 0, stream, table, vocab, hidden,
                     token, out, out2, sel, sel_value);
  return launch_status(hipGetLastError());
}

int sk_select(const int32_t* gate, int32_t gate_value, const float* a, const float* b, int32_t dim, float* out,
              hipStream_t stream) {
  if (!gate || !a || !b || !out) return SK_E_NULL;
  if (dim < 1) return SK_E_RANGE;
  hipLaunchKernelGGL(select_kernel, dim3(unsigned((dim + 255) / 256)), dim3(256), 0, stream, gate, gate_value, a, b,
                     dim, out);
  return launch_status(hipGetLastError());
}

}  // extern "C"
