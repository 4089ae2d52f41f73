// Split-K decode attention over a paged bf16 KV cache: full, local (sinks + window)
// and block-list views, with the current token's commit fused in.
//
// What is computed (per request b, query head h, KV head g = h / (Hq/Hkv), key set S):
//   o_h = sum_{j in S} softmax_j(scale * <q_h, k_{g,j}>) v_{g,j}
// with S the Full view [0, n), the Local view [0, min(s,n)) u [max(.., n-w), n)
// (On-Demand Attention summary page, "Approach"; "Main results" for the window that
// counts the current token) or the kept blocks of a Declarative-Attention keep-list
// (DA review page, section 3: block-granular mask by block-table rewrite).
//
// How (gfx950):
//  * Work item = (request, KV head, split of consecutive tiles); a tile is one
//    16-position block of one KV head (4 KiB of K and 4 KiB of V). Every workgroup
//    derives the same plan from seq_lens / selectors, so no planning launch is needed.
//  * One workgroup = 4 waves; a wave takes pairs of tiles (32 positions). K and V
//    tiles are stored in the byte order of the v_mfma_f32_16x16x32_bf16 operands, so
//    each lane issues plain coalesced 16-byte loads (1 KiB per wave instruction) that
//    are already its MFMA operand registers: no LDS staging, no shuffles.
//  * S = K q^T and O += V^T P^T run on the matrix cores. q (fp32) and p (fp32) are
//    split into bf16 hi + lo parts, so the products keep ~16 mantissa bits; the
//    accumulation is fp32. All query heads of a KV head share one read of K and V.
//  * Online softmax in base 2 (q pre-scaled by scale*log2 e), max reduced across the
//    four lane groups with shuffles; waves combine through LDS; splits are merged by
//    the last workgroup to finish (atomic ticket per (request, KV head)), in a fixed
//    split order, so results are deterministic.
#include <math.h>

#include "sk_internal.h"

namespace sk {
namespace {

enum { kFull = 0, kLocal = 1, kList = 2 };
constexpr int kMinTilesPerSplit = 2 * kWavesPerWG;  // one pair of tiles per wave
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const float* q;
  sk_paged_kv kv;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* sel;
  int sel_value;
  const int32_t* list_phys;
  const int32_t* list_cnt;
  const int32_t* list_num;
  float* out;
  int32_t* err;
  uint32_t* tickets;
  float* partials;
  int sinks;
  int window;
  float qscale;
};

struct Tile {
  int phys, lo, hi;
};

__device__ inline bool request_active(const DecodeParams& P, int b) {
  return P.sel == nullptr || P.sel[b] == P.sel_value;
}

template <int MODE>
__device__ inline int request_tiles(const DecodeParams& P, int b, int n) {
  if (MODE == kFull) return (n + kBlock - 1) / kBlock;
  if (MODE == kLocal) {
    int s_end = min(P.sinks, n);
    int a = max(s_end, n - P.window);
    int st = (s_end + kBlock - 1) / kBlock;
    int wt = (a < n) ? ((n - 1) / kBlock - a / kBlock + 1) : 0;
    return st + wt;
  }
  int k = P.list_num[b];
  return min(max(k, 0), P.kv.max_blocks);
}

template <int MODE>
__device__ inline Tile tile_at(const DecodeParams& P, int b, int n, int i) {
  Tile t;
  const int32_t* bt = P.kv.block_tables + int64_t(b) * P.kv.max_blocks;
  if (MODE == kFull) {
    t.lo = 0;
    t.hi = min(kBlock, n - kBlock * i);
    t.phys = bt[i];
  } else if (MODE == kLocal) {
    int s_end = min(P.sinks, n);
    int st = (s_end + kBlock - 1) / kBlock;
    int lb;
    if (i < st) {
      lb = i;
      t.lo = 0;
      t.hi = min(kBlock, s_end - kBlock * i);
    } else {
      int a = max(s_end, n - P.window);
      int j = i - st;
      lb = a / kBlock + j;
      t.lo = (j == 0) ? (a % kBlock) : 0;
      t.hi = min(kBlock, n - kBlock * lb);
    }
    t.phys = bt[lb];
  } else {
    int64_t o = int64_t(b) * P.kv.max_blocks + i;
    t.phys = P.list_phys[o];
    t.lo = 0;
    t.hi = min(max(P.list_cnt[o], 0), kBlock);
  }
  if (t.phys < 0 || t.phys >= P.kv.num_phys_blocks) {
    set_error(P.err, SK_DEVERR_BLOCK_ID);
    t.phys = 0;
    t.lo = t.hi = 0;
  }
  return t;
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma(u32x4 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), b, c, 0, 0, 0);
}

__device__ inline float bf16_to_f32(__bf16 x) { return float(x); }

// Writes token (n-1) of KV head g into the pool tile and returns nothing; used when
// the token's block is not attended (keep-list without it) or for invalid requests.
__device__ inline void commit_token_lanes(const DecodeParams& P, int b, int g, int n, int lane64) {
  const int Hkv = P.kv.num_kv_heads;
  int pos = n - 1;
  int phys = P.kv.block_tables[int64_t(b) * P.kv.max_blocks + pos / kBlock];
  if (phys < 0 || phys >= P.kv.num_phys_blocks) {
    set_error(P.err, SK_DEVERR_BLOCK_ID);
    return;
  }
  int t = pos % kBlock;
  size_t tile = (size_t(phys) * Hkv + g) * kTileBytes;
  uint8_t* kt = reinterpret_cast<uint8_t*>(P.kv.k_pool) + tile;
  uint8_t* vt = reinterpret_cast<uint8_t*>(P.kv.v_pool) + tile;
  const uint16_t* kn = P.k_new + (int64_t(b) * Hkv + g) * kHeadDim;
  const uint16_t* vn = P.v_new + (int64_t(b) * Hkv + g) * kHeadDim;
  if (lane64 < 16) {
    int d0 = lane64 * 8;
    *reinterpret_cast<u32x4*>(kt + (d0 >> 3) * 256 + t * 16) = *reinterpret_cast<const u32x4*>(kn + d0);
  }
  for (int d = lane64; d < kHeadDim; d += 64) {
    uint32_t off = (d >> 5) * 1024 + (t >> 2) * 256 + (d & 15) * 16 + ((d >> 4) & 1) * 8 + (t & 3) * 2;
    *reinterpret_cast<uint16_t*>(vt + off) = vn[d];
  }
}

// Replace token tl of a loaded tile (this lane's K / V operand registers) by the
// current token's key / value, and write those values into the pool tile.
__device__ inline void substitute_and_commit(const DecodeParams& P, int b, int g, int tl, int lane,
                                             uint8_t* ktile_lane, uint8_t* vtile, u32x4 (&kr)[4],
                                             u32x4 (&vr)[4]) {
  const int Hkv = P.kv.num_kv_heads;
  const int m = lane & 15, grp = lane >> 4;
  const uint16_t* kn = P.k_new + (int64_t(b) * Hkv + g) * kHeadDim;
  const uint16_t* vn = P.v_new + (int64_t(b) * Hkv + g) * kHeadDim;
  if (m == tl) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kr[c] = *reinterpret_cast<const u32x4*>(kn + 8 * (4 * c + grp));
      *reinterpret_cast<u32x4*>(ktile_lane + 1024 * c) = kr[c];
    }
  }
  if (grp == (tl >> 2)) {
    const int j = tl & 3;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t val = vn[32 * c + 16 * h + m];
        *reinterpret_cast<uint16_t*>(vtile + 1024 * c + 256 * grp + 16 * m + 8 * h + 2 * j) = uint16_t(val);
        uint32_t w = (j >> 1) ? (h ? vr[c].w : vr[c].y) : (h ? vr[c].z : vr[c].x);
        w = (j & 1) ? ((w & 0x0000FFFFu) | (val << 16)) : ((w & 0xFFFF0000u) | val);
        if (j >> 1) {
          if (h) vr[c].w = w; else vr[c].y = w;
        } else {
          if (h) vr[c].z = w; else vr[c].x = w;
        }
      }
    }
  }
}

// Zero the V halves of tokens outside [lo, hi) so that 0-weight tokens cannot bring in
// non-finite garbage (0 * NaN) through the PV product.
__device__ inline void mask_v(u32x4 (&vr)[4], int lo, int hi, int grp) {
  int t0 = 4 * grp;
  uint32_t m01 = ((t0 >= lo && t0 < hi) ? 0x0000FFFFu : 0u) | ((t0 + 1 >= lo && t0 + 1 < hi) ? 0xFFFF0000u : 0u);
  uint32_t m23 = ((t0 + 2 >= lo && t0 + 2 < hi) ? 0x0000FFFFu : 0u) | ((t0 + 3 >= lo && t0 + 3 < hi) ? 0xFFFF0000u : 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    vr[c].x &= m01;
    vr[c].y &= m23;
    vr[c].z &= m01;
    vr[c].w &= m23;
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams P) {
  constexpr int W = kWavesPerWG;
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = P.kv.batch, Hkv = P.kv.num_kv_heads, Hq = P.kv.num_q_heads, G = Hq / Hkv;
  const int maxb = P.kv.max_blocks;

  // LDS: acc [W][G][128] | m [W][16] | l [W][16] | tiles [B] | start [B+1] | misc
  float* s_acc = smem;
  float* s_m = s_acc + W * G * kHeadDim;
  float* s_l = s_m + W * 16;
  int* s_tiles = reinterpret_cast<int*>(s_l + W * 16);
  int* s_start = s_tiles + B;
  int* s_misc = s_start + B + 1;  // [0] tile sum, [1] T, [2] active requests, [3] last flag

  if (tid == 0) {
    s_misc[0] = 0;
    s_misc[2] = 0;
  }
  __syncthreads();

  // ---- plan: tiles per request (identical in every workgroup)
  {
    int my_sum = 0, my_active = 0;
    for (int b = tid; b < B; b += blockDim.x) {
      int tiles = 0;
      if (request_active(P, b)) {
        int n = P.kv.seq_lens[b];
        bool valid = n >= 1 && n <= maxb * kBlock;
        if (valid) tiles = request_tiles<MODE>(P, b, n);
        if (blockIdx.x == 0 && (!valid || tiles == 0)) {
          set_error(P.err, valid ? SK_DEVERR_EMPTY : SK_DEVERR_SEQ_LEN);
          float* o = P.out + int64_t(b) * Hq * kHeadDim;
          for (int i = 0; i < Hq * kHeadDim; ++i) o[i] = 0.f;
          if (valid && P.k_new)
            for (int g = 0; g < Hkv; ++g)
              for (int l = 0; l < 64; ++l) commit_token_lanes(P, b, g, n, l);
        }
      }
      s_tiles[b] = tiles;
      my_sum += tiles;
      my_active += tiles > 0;
    }
    if (my_sum) atomicAdd(&s_misc[0], my_sum);
    if (my_active) atomicAdd(&s_misc[2], my_active);
  }
  __syncthreads();
  if (tid == 0) {
    int total = s_misc[0];
    int budget = kTargetItems / Hkv - s_misc[2];
    if (budget < 1) budget = 1;
    int T = (total + budget - 1) / budget;
    if (T < kMinTilesPerSplit) T = kMinTilesPerSplit;
    T += T & 1;
    s_misc[1] = T;
  }
  __syncthreads();
  const int T = s_misc[1];
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < B; base += 64) {
      int b = base + lane;
      int items = (b < B) ? ((s_tiles[b] + T - 1) / T) * Hkv : 0;
      int x = items;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      if (b < B) s_start[b] = carry + x - items;
      carry += __shfl(x, 63);
    }
    if (lane == 0) s_start[B] = carry;
  }
  __syncthreads();
  const int total_items = s_start[B];

  const int ncol = lane & 15, grp = lane >> 4;
  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    // locate the request: largest b with start[b] <= item (it always has items)
    int lo_b = 0, hi_b = B - 1;
    while (lo_b < hi_b) {
      int mid = (lo_b + hi_b + 1) >> 1;
      if (s_start[mid] <= item) lo_b = mid; else hi_b = mid - 1;
    }
    const int b = lo_b;
    const int tiles_b = s_tiles[b];
    const int splits = (tiles_b + T - 1) / T;
    const int local = item - s_start[b];
    const int g = local / splits, split = local % splits;
    const int n = P.kv.seq_lens[b];
    const int t_begin = split * T, t_end = min(t_begin + T, tiles_b);
    const int npairs = (t_end - t_begin + 1) >> 1;

    // which tile receives the current token (-1: none attended here)
    int commit_tile = -1;
    const int tl = (n - 1) % kBlock;
    if (P.k_new) {
      if (MODE != kList) {
        commit_tile = tiles_b - 1;
      } else {
        int last_phys = P.kv.block_tables[int64_t(b) * maxb + (n - 1) / kBlock];
        if (P.list_phys[int64_t(b) * maxb + tiles_b - 1] == last_phys) commit_tile = tiles_b - 1;
        else if (split == 0 && wave == 0) commit_token_lanes(P, b, g, n, lane);
      }
    }

    // q of the G heads of KV head g -> MFMA B operands (hi and lo bf16 parts)
    bf16x8 qh[4], ql[4];
    {
      const float* qrow = P.q + (int64_t(b) * Hq + g * G + ncol) * kHeadDim;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[8];
        if (ncol < G) {
          f32x4 a0 = *reinterpret_cast<const f32x4*>(qrow + 8 * (4 * c + grp));
          f32x4 a1 = *reinterpret_cast<const f32x4*>(qrow + 8 * (4 * c + grp) + 4);
          x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
          x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v = x[i] * P.qscale;
          __bf16 hi = __bf16(v);
          qh[c][i] = hi;
          ql[c][i] = __bf16(v - bf16_to_f32(hi));
        }
      }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint8_t* kpool = reinterpret_cast<const uint8_t*>(P.kv.k_pool);
    const uint8_t* vpool = reinterpret_cast<const uint8_t*>(P.kv.v_pool);

    for (int p = wave; p < npairs; p += W) {
      const int i0 = t_begin + 2 * p, i1 = i0 + 1;
      const bool has1 = i1 < t_end;
      Tile T0 = tile_at<MODE>(P, b, n, i0);
      Tile T1 = has1 ? tile_at<MODE>(P, b, n, i1) : Tile{0, 0, 0};
      const size_t off0 = (size_t(T0.phys) * Hkv + g) * kTileBytes;
      const size_t off1 = (size_t(T1.phys) * Hkv + g) * kTileBytes;
      u32x4 kr0[4], vr0[4], kr1[4], vr1[4];
      if (T0.hi > T0.lo) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kr0[c] = *reinterpret_cast<const u32x4*>(kpool + off0 + 1024 * c + 16 * lane);
          vr0[c] = *reinterpret_cast<const u32x4*>(vpool + off0 + 1024 * c + 16 * lane);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) kr0[c] = vr0[c] = u32x4{0u, 0u, 0u, 0u};
      }
      if (T1.hi > T1.lo) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kr1[c] = *reinterpret_cast<const u32x4*>(kpool + off1 + 1024 * c + 16 * lane);
          vr1[c] = *reinterpret_cast<const u32x4*>(vpool + off1 + 1024 * c + 16 * lane);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) kr1[c] = vr1[c] = u32x4{0u, 0u, 0u, 0u};
      }
      if (i0 == commit_tile)
        substitute_and_commit(P, b, g, tl, lane, reinterpret_cast<uint8_t*>(P.kv.k_pool) + off0 + 16 * lane,
                              reinterpret_cast<uint8_t*>(P.kv.v_pool) + off0, kr0, vr0);
      if (has1 && i1 == commit_tile)
        substitute_and_commit(P, b, g, tl, lane, reinterpret_cast<uint8_t*>(P.kv.k_pool) + off1 + 16 * lane,
                              reinterpret_cast<uint8_t*>(P.kv.v_pool) + off1, kr1, vr1);
      if (T0.lo > 0 || T0.hi < kBlock) mask_v(vr0, T0.lo, T0.hi, grp);
      if (T1.lo > 0 || T1.hi < kBlock) mask_v(vr1, T1.lo, T1.hi, grp);

      // S = K q^T for both tiles: lane holds tokens 4*grp + j of head ncol
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s0 = mfma(kr0[c], qh[c], s0);
        s0 = mfma(kr0[c], ql[c], s0);
        s1 = mfma(kr1[c], qh[c], s1);
        s1 = mfma(kr1[c], ql[c], s1);
      }
      float sv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int t = 4 * grp + j;
        sv[j] = (t >= T0.lo && t < T0.hi) ? s0[j] : -INFINITY;
        sv[4 + j] = (t >= T1.lo && t < T1.hi) ? s1[j] : -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float pv[8], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
        psum += pv[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 hi = __bf16(pv[j]);
        ph[j] = hi;
        pl[j] = __bf16(pv[j] - bf16_to_f32(hi));
      }
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const int c = dc >> 1;
        u32x4 a = (dc & 1) ? u32x4{vr0[c].z, vr0[c].w, vr1[c].z, vr1[c].w}
                           : u32x4{vr0[c].x, vr0[c].y, vr1[c].x, vr1[c].y};
        acc[dc] *= alpha;
        acc[dc] = mfma(a, ph, acc[dc]);
        acc[dc] = mfma(a, pl, acc[dc]);
      }
    }

    // ---- combine the waves of this workgroup
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (ncol < G) {
#pragma unroll
      for (int dc = 0; dc < 8; ++dc)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_acc[(wave * G + ncol) * kHeadDim + 16 * dc + 4 * grp + j] = acc[dc][j];
      if (grp == 0) {
        s_m[wave * 16 + ncol] = m_run;
        s_l[wave * 16 + ncol] = l_run;
      }
    }
    __syncthreads();
    float* part = P.partials + size_t(item) * G * (kHeadDim + 2);
    for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
      const int h = idx >> 7, d = idx & (kHeadDim - 1);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w * 16 + h]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        float e = __builtin_amdgcn_exp2f(s_m[w * 16 + h] - Mu);
        L += s_l[w * 16 + h] * e;
        A += s_acc[(w * G + h) * kHeadDim + d] * e;
      }
      if (splits == 1) {
        P.out[(int64_t(b) * Hq + g * G + h) * kHeadDim + d] = (L > 0.f) ? A / L : 0.f;
      } else {
        part[h * kHeadDim + d] = A;
        if (d == 0) {
          part[G * kHeadDim + h] = M;
          part[G * (kHeadDim + 1) + h] = L;
        }
      }
    }

    // ---- the last split of (b, g) to finish merges all splits
    if (splits > 1) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        unsigned prev = atomicAdd(&P.tickets[b * Hkv + g], 1u);
        s_misc[3] = (prev == unsigned(splits - 1));
      }
      __syncthreads();
      if (s_misc[3]) {
        __threadfence();
        const int item0 = s_start[b] + g * splits;
        const size_t stride = size_t(G) * (kHeadDim + 2);
        const float* base = P.partials + size_t(item0) * stride;
        for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
          const int h = idx >> 7, d = idx & (kHeadDim - 1);
          float M = -INFINITY;
          for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * stride + G * kHeadDim + h]);
          const float Mu = (M == -INFINITY) ? 0.f : M;
          float L = 0.f, A = 0.f;
          for (int s = 0; s < splits; ++s) {
            const float* ps = base + s * stride;
            float e = __builtin_amdgcn_exp2f(ps[G * kHeadDim + h] - Mu);
            L += ps[G * (kHeadDim + 1) + h] * e;
            A += ps[h * kHeadDim + d] * e;
          }
          P.out[(int64_t(b) * Hq + g * G + h) * kHeadDim + d] = (L > 0.f) ? A / L : 0.f;
        }
        if (tid == 0) P.tickets[b * Hkv + g] = 0u;
      }
    }
    __syncthreads();
  }
}

// Keep-mask -> ascending list of (physical block, valid positions). One workgroup per
// request; block-wide exclusive scan of per-thread popcounts keeps the order.
__global__ __launch_bounds__(256) void gather_kernel(sk_paged_kv kv, const uint32_t* __restrict__ mask,
                                                     const int32_t* __restrict__ sel, int sel_value,
                                                     int32_t* __restrict__ gathered, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ num_kept, int32_t* err) {
  __shared__ int s_wave[4];
  __shared__ int s_base;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (sel && sel[b] != sel_value) return;
  const int n = kv.seq_lens[b];
  const int maxb = kv.max_blocks;
  const int words_row = (maxb + 31) / 32;
  if (n < 1 || n > maxb * kBlock) {
    if (tid == 0) {
      num_kept[b] = 0;
      set_error(err, SK_DEVERR_SEQ_LEN);
    }
    return;
  }
  const int nb = (n + kBlock - 1) / kBlock;
  const int words = (nb + 31) / 32;
  const uint32_t* mrow = mask + int64_t(b) * words_row;
  const int32_t* bt = kv.block_tables + int64_t(b) * maxb;
  int32_t* grow = gathered + int64_t(b) * maxb;
  int32_t* crow = cnt + int64_t(b) * maxb;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int w0 = 0; w0 < words; w0 += blockDim.x) {
    const int w = w0 + tid;
    uint32_t bits = 0u;
    if (w < words) {
      bits = mrow[w];
      int valid = nb - 32 * w;  // blocks of this word below nb
      if (valid < 32) bits &= (1u << valid) - 1u;
    }
    int c = __popc(bits);
    int x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < wave; ++i) wbase += s_wave[i];
    int pos = s_base + wbase + x - c;
    while (bits) {
      int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      int blk = 32 * w + bit;
      grow[pos] = bt[blk];
      crow[pos] = min(kBlock, n - kBlock * blk);
      ++pos;
    }
    __syncthreads();
    if (tid == 0) s_base += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
  }
  if (tid == 0) num_kept[b] = s_base;
}

template <int MODE>
int launch_decode(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int sinks, int window,
                  float scale, const int32_t* sel, int sel_value, const int32_t* lp, const int32_t* lc,
                  const int32_t* ln, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!q || !out || !ws) return SK_E_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return SK_E_NULL;
  if (ws_bytes < sk_workspace_bytes(kv.batch, kv.num_q_heads)) return SK_E_WORKSPACE;
  DecodeParams P;
  P.q = q;
  P.kv = kv;
  P.k_new = reinterpret_cast<const uint16_t*>(k_new);
  P.v_new = reinterpret_cast<const uint16_t*>(v_new);
  P.sel = sel;
  P.sel_value = sel_value;
  P.list_phys = lp;
  P.list_cnt = lc;
  P.list_num = ln;
  P.out = out;
  P.err = reinterpret_cast<int32_t*>(ws);
  P.tickets = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + kWsHeaderBytes);
  P.partials = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + kPartialsOffset);
  P.sinks = sinks;
  P.window = window;
  P.qscale = scale * kLog2e;
  const int G = kv.num_q_heads / kv.num_kv_heads;
  // upper bound of the work items, so that tiny launches do not dispatch idle workgroups
  int64_t tiles_max = (MODE == kLocal)
                          ? int64_t((sinks + kBlock - 1) / kBlock) + (window + kBlock - 1) / kBlock + 1
                          : int64_t(kv.max_blocks);
  if (tiles_max > kv.max_blocks) tiles_max = kv.max_blocks;
  int64_t bound = int64_t(kv.batch) * kv.num_kv_heads * ((tiles_max + kMinTilesPerSplit - 1) / kMinTilesPerSplit);
  int grid = int(bound < kTargetItems ? bound : kTargetItems);
  if (grid < 1) grid = 1;
  size_t lds = size_t(kWavesPerWG) * G * kHeadDim * 4 + size_t(kWavesPerWG) * 16 * 4 * 2 +
               size_t(2 * kv.batch + 1 + 4) * 4;
  hipLaunchKernelGGL(decode_kernel<MODE>, dim3(grid), dim3(64 * kWavesPerWG), lds, stream, P);
  return launch_status(hipGetLastError());
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int oda_decode_local(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int32_t sinks,
                     int32_t window, float scale, const int32_t* sel, int32_t sel_value, float* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  return launch_decode<kLocal>(q, kv, k_new, v_new, sinks, window, scale, sel, sel_value, nullptr, nullptr,
                               nullptr, out, ws, ws_bytes, stream);
}

int oda_decode_full(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, float scale,
                    const int32_t* sel, int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return launch_decode<kFull>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, nullptr, nullptr, nullptr, out,
                              ws, ws_bytes, stream);
}

int da_decode_blocks(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                     const uint32_t* keep_mask, int32_t* gathered, int32_t* gathered_cnt, int32_t* num_kept,
                     float scale, const int32_t* sel, int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!keep_mask || !gathered || !gathered_cnt || !num_kept || !ws) return SK_E_NULL;
  hipLaunchKernelGGL(gather_kernel, dim3(kv.batch), dim3(256), 0, stream, kv, keep_mask, sel, sel_value, gathered,
                     gathered_cnt, num_kept, reinterpret_cast<int32_t*>(ws));
  st = launch_status(hipGetLastError());
  if (st) return st;
  return launch_decode<kList>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, gathered, gathered_cnt, num_kept,
                              out, ws, ws_bytes, stream);
}

}  // extern "C"
