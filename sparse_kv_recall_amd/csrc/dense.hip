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
// whole output rows and walks them with a two-deep register ring: the next row's 16-byte
// weight loads are in flight while this row is reduced; loads past the last row go
// through an empty buffer range (zeros, no memory access), so the loop has no branches.
// The workgroup stages the input vector in LDS once (RMSNorm prologue, fp32), lanes
// form partial dot products, and a DPP wave reduction sums them in a fixed order
// (deterministic). Residual add and the SwiGLU product (gate and up rows paired in one
// wave) are fused into the store. The q/k/v projection is one such GEMV followed by a
// per-head kernel for the q/k RMS norm and the rotary pairs (i, i + 64), with rotary
// angles computed in fp64 (sk_qkv_rope); the decode launches can instead apply that
// per-head finish themselves to the GEMV's raw output (oda_decode_*_qkv, decode.hip).
// Each thread requests its share of the input vector before the weights: loads complete
// in issue order, so the wait for the input then leaves the weight loads in flight.
#include <math.h>

#include "sk_internal.h"

namespace sk {
namespace {

constexpr int kGemvWaves = 8;   // waves per GEMV workgroup
constexpr int kGemvGrid = 512;  // GEMV workgroups at most (two per CU)

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

// The thread's share of the input vector (cols = 512 J floats, 512 threads): elements
// t + 512 j, j < J, and their RMSNorm gains. Requested before the weights, so that the
// wait for them leaves the weight loads in flight: the loads of a wave complete in issue
// order, and a staging loop issued after the weights would wait for them on every
// iteration.
template <int J, int PRO>
__device__ inline void load_input(const float* __restrict__ x, const uint16_t* __restrict__ gamma, float (&xv)[J],
                                  float (&gv)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) xv[j] = x[threadIdx.x + 512 * j];
  if (PRO == SK_PRO_RMSNORM) {
#pragma unroll
    for (int j = 0; j < J; ++j) gv[j] = bf16f(gamma[threadIdx.x + 512 * j]);
  }
}

// Stage the prologue's input vector in LDS (RMSNorm over all cols values when PRO asks).
template <int J, int PRO>
__device__ inline void stage_input(const float (&xv)[J], const float (&gv)[J], float eps, float* xs, float* red) {
  if (PRO == SK_PRO_RMSNORM) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) ss = fmaf(xv[j], xv[j], ss);
    const float r = 1.f / sqrtf(block_sum(ss, red) / float(512 * J) + eps);
#pragma unroll
    for (int j = 0; j < J; ++j) xs[threadIdx.x + 512 * j] = xv[j] * r * gv[j];
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) xs[threadIdx.x + 512 * j] = xv[j];
  }
  __syncthreads();
}

// A wave-uniform address in scalar registers (buffer resources must be uniform).
__device__ inline const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return reinterpret_cast<const uint8_t*>((uint64_t(hi) << 32) | lo);
}

constexpr int kBufferFlags = 0x00020000;  // raw buffer access, 32-bit data format (gfx9 word 3)
constexpr int kNonTemporal = 2;

// The lane's J 16-byte chunks of one weight row, through a buffer resource spanning the
// row: when ok is false the range is empty and the loads return zeros without touching
// memory, so fetches past the last row need no branch.
template <int J>
__device__ inline void load_row(const uint16_t* W, int row, int cols, bool ok, int lane, u32x4 (&w)[J]) {
  const uint8_t* base = uniform_ptr(reinterpret_cast<const uint8_t*>(W) + size_t(row) * cols * 2);
  const int bytes = __builtin_amdgcn_readfirstlane(ok ? cols * 2 : 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kBufferFlags);
#pragma unroll
  for (int j = 0; j < J; ++j)
    w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (lane + 64 * j), 0, kNonTemporal));
}

// residual[row], or 0 when there is no residual or no row: one unconditional load through
// a buffer range that is empty in those cases (no memory access), so that the number of
// loads in flight, which the waits count, does not depend on a branch.
__device__ inline float load_residual(const float* residual, int rows, int row, bool ok) {
  const int bytes = residual ? rows * 4 : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(residual), 0, bytes, kBufferFlags);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? row * 4 : bytes, 0, 0));
}

template <int J>
__device__ inline float row_dot(const u32x4 (&w)[J], const float* xs, int lane) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) acc += dot8(w[j], xs + 8 * (lane + 64 * j));
  return wave_sum(acc);
}

// Persistent GEMV: every wave walks the output rows g, g + G, ... (G = waves in the
// grid) with a two-deep register ring, so the next row's weights are in flight while
// this row is reduced. EPI_SWIGLU pairs weight rows r (gate) and rows + r (up) in one
// wave and stores SiLU(gate) * up.
template <int J, int PRO, int EPI>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_kernel(const uint16_t* __restrict__ W, int rows, int cols,
                                                               const float* __restrict__ x,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               const float* residual, float* y, const int32_t* sel,
                                                               int sel_value) {
  constexpr int NR = (EPI == SK_EPI_SWIGLU) ? 2 : 1;
  constexpr bool kRing = NR * J <= 12;  // two row buffers fit the registers
  if (gated_off(sel, sel_value)) return;
  extern __shared__ float xs[];
  __shared__ float red[kGemvWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = int(gridDim.x) * kGemvWaves;
  int it = int(blockIdx.x) * kGemvWaves + wave;
  float xv[J], gv[J];
  load_input<J, PRO>(x, gamma, xv, gv);
  u32x4 b0[NR][J], b1[NR][J];  // b1 is only used (and allocated) with the ring
  float r0 = 0.f, r1 = 0.f;     // the residuals of the rows in b0 / b1
  // A row's weights and its residual are requested together.
  auto fetch = [&](u32x4 (&b)[NR][J], float& res, int item) {
    const bool ok = item < rows;
    const int r = ok ? item : 0;
#pragma unroll
    for (int k = 0; k < NR; ++k) load_row<J>(W, r + k * rows, cols, ok, lane, b[k]);
    if (EPI != SK_EPI_SWIGLU) res = load_residual(residual, rows, r, ok);
  };
  auto finish = [&](u32x4 (&b)[NR][J], float res, int item) {
    const float a0 = row_dot<J>(b[0], xs, lane);
    float v;
    if (EPI == SK_EPI_SWIGLU) {
      const float a1 = row_dot<J>(b[NR - 1], xs, lane);
      v = a0 / (1.f + expf(-a0)) * a1;
    } else {
      v = a0 + res;
    }
    if (lane == 0) y[item] = v;
  };
  fetch(b0, r0, it);
  stage_input<J, PRO>(xv, gv, eps, xs, red);
  if constexpr (kRing) {
    for (; it + G < rows; it += 2 * G) {
      fetch(b1, r1, it + G);
      finish(b0, r0, it);
      fetch(b0, r0, it + 2 * G);
      finish(b1, r1, it + G);
    }
    if (it < rows) finish(b0, r0, it);
  } else {  // wide rows: one row (pair) in flight per wave, the other waves overlap it
    finish(b0, r0, it);
    for (it += G; it < rows; it += G) {
      fetch(b0, r0, it);
      finish(b0, r0, it);
    }
  }
}

// Per-head tail of the q/k/v projection: q and k heads RMS-normalised over their 128
// values and rotated (RoPE, pairs (i, i + 64), angles in fp64); k and v rounded to bf16.
__global__ __launch_bounds__(kHeadDim) void qk_finish_kernel(const float* __restrict__ raw,
                                                            const uint16_t* __restrict__ g_q,
                                                            const uint16_t* __restrict__ g_k, int Hq, int Hkv,
                                                            float eps, float rope_base,
                                                            const int32_t* __restrict__ seq_lens, float* q_out,
                                                            uint16_t* k_out, uint16_t* v_out, const int32_t* sel,
                                                            int sel_value) {
  __shared__ float red[kHeadDim / 64];
  __shared__ float s_val[kHeadDim];
  if (gated_off(sel, sel_value)) return;
  const int head = blockIdx.x, t = threadIdx.x;
  const bool is_q = head < Hq, is_v = head >= Hq + Hkv;
  float v = raw[head * kHeadDim + t];
  // the gain is requested with the projection row, not after the reduction's barriers
  // (v heads read a k gain they do not use, so the load needs no branch)
  const uint16_t gain = (is_q ? g_q : g_k)[t];
  // rotary angle of pair t % 64 at position n - 1, in fp64 and reduced to [-pi, pi]
  // before the sine and cosine (|angle| < 2^31 rad, so the reduction error stays far
  // below fp32 resolution); computed while the projection row is still loading
  float c = 1.f, s = 0.f;
  if (!is_v) {
    const int i = t & 63;
    const double ang = double(seq_lens[0] - 1) * exp2(-double(i) / 64.0 * log2(double(rope_base)));
    const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    double sd, cd;
    sincos(red, &sd, &cd);
    c = float(cd);
    s = float(sd);
  }
  const float ss = block_sum(v * v, red);
  if (!is_v) v = v * (1.f / sqrtf(ss / float(kHeadDim) + eps)) * bf16f(gain);
  s_val[t] = v;
  __syncthreads();
  float o = v;
  if (!is_v) o = (t < 64) ? v * c - s_val[t + 64] * s : v * c + s_val[t - 64] * s;
  if (is_q) {
    q_out[head * kHeadDim + t] = o;
  } else {
    uint16_t* dst = is_v ? v_out + (head - Hq - Hkv) * kHeadDim : k_out + (head - Hq) * kHeadDim;
    dst[t] = __builtin_bit_cast(uint16_t, __bf16(o));
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

template <int J>
int launch_gemv_j(const uint16_t* W, int rows, int cols, const float* x, int pro, int epi, const uint16_t* gamma,
                  float eps, const float* residual, float* y, const int32_t* sel, int sel_value, hipStream_t stream) {
  const int waves = rows;  // one output row (pair) per wave while the grid allows
  int wgs = (waves + kGemvWaves - 1) / kGemvWaves;
  if (wgs > kGemvGrid) wgs = kGemvGrid;
  const dim3 grid{unsigned(wgs)}, block{unsigned(64 * kGemvWaves)};
  const size_t lds = size_t(cols) * 4;
#define SK_GEMV(P, E)                                                                                             \
  hipLaunchKernelGGL((gemv_kernel<J, P, E>), grid, block, lds, stream, W, rows, cols, x, gamma, eps, residual, y, \
                     sel, sel_value)
  if (pro == SK_PRO_RMSNORM) {
    if (epi == SK_EPI_SWIGLU) SK_GEMV(SK_PRO_RMSNORM, SK_EPI_SWIGLU);
    else SK_GEMV(SK_PRO_RMSNORM, SK_EPI_STORE);
  } else {
    if (epi == SK_EPI_SWIGLU) SK_GEMV(SK_PRO_NONE, SK_EPI_SWIGLU);
    else SK_GEMV(SK_PRO_NONE, SK_EPI_STORE);
  }
#undef SK_GEMV
  return launch_status(hipGetLastError());
}

int launch_gemv(const uint16_t* W, int rows, int cols, const float* x, int pro, int epi, const uint16_t* gamma,
                float eps, const float* residual, float* y, const int32_t* sel, int sel_value, hipStream_t stream) {
  switch (cols / 512) {
#define SK_J(JJ) \
  case JJ: return launch_gemv_j<JJ>(W, rows, cols, x, pro, epi, gamma, eps, residual, y, sel, sel_value, stream);
    SK_J(1)
    SK_J(2)
    SK_J(3)
    SK_J(4)
    SK_J(6)
    SK_J(8)
    SK_J(12)
    SK_J(16)
#undef SK_J
    default: return SK_E_SHAPE;
  }
}

bool valid_width(int cols) { return cols >= 512 && cols <= 8192 && cols % 512 == 0; }

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_gemv(const uint16_t* W, int32_t rows, int32_t cols, const float* x, int32_t prologue, const uint16_t* gamma,
            float eps, const float* residual, int32_t epilogue, float* y, const int32_t* sel, int32_t sel_value,
            hipStream_t stream) {
  if (!W || !x || !y) return SK_E_NULL;
  if (prologue < SK_PRO_NONE || prologue > SK_PRO_RMSNORM || rows < 1) return SK_E_RANGE;
  if (epilogue < SK_EPI_STORE || epilogue > SK_EPI_SWIGLU) return SK_E_RANGE;
  if (epilogue == SK_EPI_SWIGLU && residual) return SK_E_RANGE;
  if (prologue == SK_PRO_RMSNORM && !gamma) return SK_E_NULL;
  if (!valid_width(cols)) return SK_E_SHAPE;
  if (x == y) return SK_E_RANGE;
  return launch_gemv(W, rows, cols, x, prologue, epilogue, gamma, eps, residual, y, sel, sel_value, stream);
}

int sk_qkv_rope(const uint16_t* W_qkv, const float* h, const uint16_t* g_attn, const uint16_t* g_q,
                const uint16_t* g_k, int32_t hidden, int32_t q_heads, int32_t kv_heads, float eps, float rope_base,
                const int32_t* seq_lens, float* scratch, float* q_out, uint16_t* k_out, uint16_t* v_out,
                const int32_t* sel, int32_t sel_value, hipStream_t stream) {
  if (!W_qkv || !h || !g_attn || !g_q || !g_k || !seq_lens || !scratch || !q_out || !k_out || !v_out)
    return SK_E_NULL;
  if (kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0) return SK_E_HEADS;
  if (q_heads + 2 * kv_heads > 65535 || !(rope_base > 0.f)) return SK_E_RANGE;
  if (!valid_width(hidden)) return SK_E_SHAPE;
  const int heads = q_heads + 2 * kv_heads;
  int st = launch_gemv(W_qkv, heads * kHeadDim, hidden, h, SK_PRO_RMSNORM, SK_EPI_STORE, g_attn, eps, nullptr,
                       scratch, sel, sel_value, stream);
  if (st) return st;
  hipLaunchKernelGGL(qk_finish_kernel, dim3(unsigned(heads)), dim3(kHeadDim), 0, stream, scratch, g_q, g_k, q_heads,
                     kv_heads, eps, rope_base, seq_lens, q_out, k_out, v_out, sel, sel_value);
  return launch_status(hipGetLastError());
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
